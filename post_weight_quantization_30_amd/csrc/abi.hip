// abi.hip -- the extern "C" entry points of libawq.so (declared in include/awq.h).
//
// Every entry point validates all arguments on the host before it enqueues
// anything; on a failed check it returns a negative status and writes nothing.
// The library allocates no device memory: scratch comes from the caller's
// workspace, or for awq_search_noalloc from a static device array.
#include <mutex>

#include "awq_internal.h"

namespace {

bool valid_dtype(int d) { return d == AWQ_F32 || d == AWQ_F16 || d == AWQ_BF16; }
bool valid_mode(int m) { return m == AWQ_SYM || m == AWQ_ASYM; }

int hip_status(hipError_t e) { return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP; }

bool search_group_ok(int g) { return g == 32 || g == 64 || g == 128; }
bool pack_group_ok(int g)
{
    return g == 32 || g == 64 || g == 128 || g == 256 || g == 512 || g == 1024 || g == 2048;
}

}  // namespace

extern "C" {

const char *awq_status_string(int status)
{
    switch (status) {
    case AWQ_OK: return "ok";
    case AWQ_ERR_INVALID_ARG: return "invalid argument";
    case AWQ_ERR_WORKSPACE: return "workspace too small";
    case AWQ_ERR_HIP: return "HIP runtime error";
    case AWQ_ERR_NONFINITE: return "no finite candidate error";
    case AWQ_ERR_UNSUPPORTED: return "unsupported by the GPU kernels";
    default: return "unknown status";
    }
}

size_t awq_act_stats_workspace_size(int64_t tokens, int64_t in)
{
    (void)tokens;
    (void)in;
    return 0;   // the statistics kernel keeps its partial sums in LDS
}

int awq_act_stats(const void *X, int dtype, int64_t tokens, int64_t in, float *xmag, void *ws,
                  size_t ws_bytes, void *stream)
{
    if (!X || !xmag || tokens < 1 || in < 1 || !valid_dtype(dtype))
        return AWQ_ERR_INVALID_ARG;
    (void)ws;
    (void)ws_bytes;
    if ((in + 63) / 64 > (int64_t)0x7fffffff)
        return AWQ_ERR_UNSUPPORTED;
    return hip_status(awq::launch_act_stats(X, dtype, tokens, in, xmag, (hipStream_t)stream));
}

int awq_s_table(const float *xmag, int64_t in, int grid, float *s_table, void *stream)
{
    if (!xmag || !s_table || in < 1 || grid < 1 || grid > AWQ_MAX_GRID)
        return AWQ_ERR_INVALID_ARG;
    if ((in + 255) / 256 > (int64_t)0x7fffffff)
        return AWQ_ERR_UNSUPPORTED;
    return hip_status(awq::launch_s_table(xmag, in, grid, s_table, nullptr, nullptr,
                                          (hipStream_t)stream));
}

size_t awq_search_workspace_size(int64_t out, int64_t in, int64_t tokens, int grid)
{
    if (out < 1 || in < 1 || tokens < 1 || grid < 1 || grid > AWQ_MAX_GRID)
        return 0;
    return awq::search_ws_layout(out, in, tokens, grid).total;
}

namespace {

// The search, clipping and packing kernels read W, X, s and the workspace in
// 16-byte vectors: their base addresses must be 16-byte aligned (any
// allocation is; an offset view need not be).
bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_search_shape(int64_t out, int64_t in, int64_t tokens, int grid)
{
    if (out < 1 || in < 1 || tokens < 1 || grid < 1 || grid > AWQ_MAX_GRID)
        return AWQ_ERR_INVALID_ARG;
    return AWQ_OK;
}

int check_workspace(int64_t out, int64_t in, int64_t tokens, int grid, const void *ws,
                    size_t ws_bytes, awq::SearchWs *lay)
{
    *lay = awq::search_ws_layout(out, in, tokens, grid);
    if (!ws || ws_bytes < lay->total)
        return AWQ_ERR_WORKSPACE;
    if (!aligned16(ws))
        return AWQ_ERR_UNSUPPORTED;
    if (lay->nblk > (int64_t)0x7fffffff || (tokens + awq::kTokPerBlock - 1) / awq::kTokPerBlock > 65535 ||
        (in + 255) / 256 > (int64_t)0x7fffffff)
        return AWQ_ERR_UNSUPPORTED;
    return AWQ_OK;
}

int check_candidates(const void *W, const void *X, int dtype, int64_t in, int bits, int group,
                     int mode)
{
    if (!W || !X || group < 1 || in % group != 0 || bits < 2 || bits > 8 || !valid_dtype(dtype) ||
        !valid_mode(mode))
        return AWQ_ERR_INVALID_ARG;
    if (!aligned16(W) || !aligned16(X))
        return AWQ_ERR_UNSUPPORTED;
    return AWQ_OK;
}

}  // namespace

int awq_search_prepare(const void *X, int dtype, const float *xmag, int64_t out, int64_t in,
                       int64_t tokens, int grid, void *ws, size_t ws_bytes, void *stream)
{
    if (!X || !xmag || !valid_dtype(dtype))
        return AWQ_ERR_INVALID_ARG;
    int st = check_search_shape(out, in, tokens, grid);
    awq::SearchWs lay;
    if (st == AWQ_OK)
        st = check_workspace(out, in, tokens, grid, ws, ws_bytes, &lay);
    if (st == AWQ_OK && !aligned16(X))
        st = AWQ_ERR_UNSUPPORTED;
    if (st != AWQ_OK)
        return st;
    char *base = (char *)ws;
    return hip_status(awq::launch_prepare(X, dtype, xmag, out, in, tokens, grid, (float *)(base + lay.s_off),
                                          (float *)(base + lay.inv_off), (int32_t *)(base + lay.unit_off),
                                          base + lay.xf_off, (hipStream_t)stream));
}

int awq_search_candidates(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                          int64_t tokens, int bits, int group, int grid, int mode, void *ws,
                          size_t ws_bytes, void *stream)
{
    int st = check_candidates(W, X, dtype, in, bits, group, mode);
    if (st == AWQ_OK)
        st = check_search_shape(out, in, tokens, grid);
    awq::SearchWs lay;
    if (st == AWQ_OK)
        st = check_workspace(out, in, tokens, grid, ws, ws_bytes, &lay);
    if (st == AWQ_OK && !search_group_ok(group))
        st = AWQ_ERR_UNSUPPORTED;
    if (st != AWQ_OK)
        return st;
    char *base = (char *)ws;
    return hip_status(awq::launch_search(W, X, dtype, out, in, tokens, (const float *)(base + lay.s_off),
                                         (const float *)(base + lay.inv_off),
                                         (const int32_t *)(base + lay.unit_off), grid + 1, bits,
                                         group, mode, (double *)(base + lay.part_off),
                                         base + lay.xf_off, nullptr, (hipStream_t)stream));
}

int awq_search_finish(int64_t out, int64_t in, int64_t tokens, int grid, double *mse,
                      int32_t *best, float *s_best, void *ws, size_t ws_bytes, void *stream)
{
    if (!mse || !best || !s_best)
        return AWQ_ERR_INVALID_ARG;
    int st = check_search_shape(out, in, tokens, grid);
    awq::SearchWs lay;
    if (st == AWQ_OK)
        st = check_workspace(out, in, tokens, grid, ws, ws_bytes, &lay);
    if (st != AWQ_OK)
        return st;
    char *base = (char *)ws;
    return hip_status(awq::launch_reduce_argmin((const double *)(base + lay.part_off), lay.nblk,
                                                grid + 1, out, tokens, in,
                                                (const float *)(base + lay.s_off), mse, best,
                                                s_best, (hipStream_t)stream));
}

// The single call: the three stages, validated together up front and
// enqueued back to back.
int awq_search(const void *W, const void *X, int dtype, int64_t out, int64_t in, int64_t tokens,
               const float *xmag, int bits, int group, int grid, int mode, double *mse,
               int32_t *best, float *s_best, void *ws, size_t ws_bytes, void *stream)
{
    // Validate everything for all stages before the first launch.
    if (!xmag || !mse || !best || !s_best)
        return AWQ_ERR_INVALID_ARG;
    int st = check_candidates(W, X, dtype, in, bits, group, mode);
    if (st == AWQ_OK)
        st = check_search_shape(out, in, tokens, grid);
    awq::SearchWs lay;
    if (st == AWQ_OK)
        st = check_workspace(out, in, tokens, grid, ws, ws_bytes, &lay);
    if (st == AWQ_OK && !search_group_ok(group))
        st = AWQ_ERR_UNSUPPORTED;
    if (st != AWQ_OK)
        return st;
    st = awq_search_prepare(X, dtype, xmag, out, in, tokens, grid, ws, ws_bytes, stream);
    if (st != AWQ_OK)
        return st;
    char *base = (char *)ws;
    const awq::FinishOut fin{mse, best, s_best};
    return hip_status(awq::launch_search(W, X, dtype, out, in, tokens, (const float *)(base + lay.s_off),
                                         (const float *)(base + lay.inv_off),
                                         (const int32_t *)(base + lay.unit_off), grid + 1, bits,
                                         group, mode, (double *)(base + lay.part_off),
                                         base + lay.xf_off, &fin, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Scratch of awq_search_noalloc. Every GPU the library runs on holds its own
// copy until the process ends. In host code `scratch` only names the symbol:
// its device address, different on each GPU, comes from hipGetSymbolAddress
// with that GPU current, and only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[AWQ_SEARCH_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch, looked up once per device.
int current_scratch(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return AWQ_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices)
        return AWQ_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return AWQ_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return AWQ_OK;
}

}  // namespace

extern "C" {

int awq_search_noalloc(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                       int64_t tokens, const float *xmag, int bits, int group, int grid, int mode,
                       double *mse, int32_t *best, float *s_best, void *stream)
{
    // Shape and size checks first: a refused call touches no device.
    int st = check_search_shape(out, in, tokens, grid);
    if (st != AWQ_OK)
        return st;
    if (awq::search_ws_layout(out, in, tokens, grid).total > AWQ_SEARCH_NOALLOC_MAX_BYTES)
        return AWQ_ERR_WORKSPACE;
    if (!W || !X || !xmag || !mse || !best || !s_best)
        return AWQ_ERR_INVALID_ARG;
    void *ws = nullptr;
    st = current_scratch(&ws);
    if (st != AWQ_OK)
        return st;
    return awq_search(W, X, dtype, out, in, tokens, xmag, bits, group, grid, mode, mse, best,
                      s_best, ws, AWQ_SEARCH_NOALLOC_MAX_BYTES, stream);
}

int awq_quantize_pack(const void *W, int dtype, int64_t out, int64_t in, const float *s, int bits,
                      int group, int mode, uint32_t *qweight, float *scales, uint8_t *zeros,
                      void *stream)
{
    return awq_quantize_pack_clip(W, dtype, out, in, s, nullptr, bits, group, mode, qweight, scales,
                                  zeros, stream);
}

namespace {

int fold_call(const void *A, int dtype, int64_t rows, int64_t cols, const float *s, void *out,
              bool scale_cols, void *stream)
{
    if (!A || !s || !out || rows < 1 || cols < 1 || !valid_dtype(dtype))
        return AWQ_ERR_INVALID_ARG;
    if (rows > INT64_MAX / cols)
        return AWQ_ERR_INVALID_ARG;
    return hip_status(awq::launch_fold(A, dtype, rows, cols, s, out, scale_cols, (hipStream_t)stream));
}

}  // namespace

int awq_fold_rows(const void *A, int dtype, int64_t rows, int64_t cols, const float *s, void *out,
                  void *stream)
{
    return fold_call(A, dtype, rows, cols, s, out, false, stream);
}

int awq_scale_cols(const void *W, int dtype, int64_t rows, int64_t cols, const float *s, void *out,
                   void *stream)
{
    return fold_call(W, dtype, rows, cols, s, out, true, stream);
}

size_t awq_gptq_factor_workspace_size(int64_t in)
{
    if (in < 1)
        return 0;
    return awq::align256((size_t)(in * in + (in * in + 3) / 4) * sizeof(double));
}

size_t awq_gptq_quantize_workspace_size(int64_t out, int64_t in)
{
    if (out < 1 || in < 1)
        return 0;
    return awq::align256((size_t)(out * in + out * 128) * sizeof(double));
}

size_t awq_gptq_workspace_size(int64_t out, int64_t in)
{
    if (out < 1 || in < 1)
        return 0;
    const size_t f = awq_gptq_factor_workspace_size(in), q = awq_gptq_quantize_workspace_size(out, in);
    return 2 * awq::align256((size_t)(in * in) * sizeof(double)) + (f > q ? f : q);
}

namespace {

int gptq_shape(int64_t in)
{
    if (in < 1)
        return AWQ_ERR_INVALID_ARG;
    if (in % 128 != 0 || in > 65535LL * 64)
        return AWQ_ERR_UNSUPPORTED;
    return AWQ_OK;
}

}  // namespace

int awq_gptq_hessian(const void *X, int dtype, int64_t tokens, int64_t in, double damp, double *H,
                     void *stream)
{
    if (!X || !H || tokens < 1 || !valid_dtype(dtype) || !(damp >= 0.0 && damp < 1e300))
        return AWQ_ERR_INVALID_ARG;
    int st = gptq_shape(in);
    if (st != AWQ_OK)
        return st;
    return hip_status(awq::launch_gptq_hessian(X, dtype, tokens, in, damp, H, (hipStream_t)stream));
}

int awq_gptq_factor(const double *H, int64_t in, double *U, void *ws, size_t ws_bytes, void *stream)
{
    if (!H || !U)
        return AWQ_ERR_INVALID_ARG;
    int st = gptq_shape(in);
    if (st != AWQ_OK)
        return st;
    if (!ws || ws_bytes < awq_gptq_factor_workspace_size(in))
        return AWQ_ERR_WORKSPACE;
    return hip_status(awq::launch_gptq_factor(H, in, U, (double *)ws, (hipStream_t)stream));
}

int awq_gptq_quantize(const void *W, int dtype, int64_t out, int64_t in, const double *U, int bits,
                      int group, int mode, uint32_t *qweight, float *scales, uint8_t *zeros, void *ws,
                      size_t ws_bytes, void *stream)
{
    if (!W || !U || !qweight || !scales || !zeros || out < 1 || group < 1 || in % group != 0 ||
        bits < 2 || bits > 8 || !valid_dtype(dtype) || !valid_mode(mode))
        return AWQ_ERR_INVALID_ARG;
    int st = gptq_shape(in);
    if (st != AWQ_OK)
        return st;
    if (!search_group_ok(group) || (out + 3) / 4 > (int64_t)0x7fffffff || out > 65535LL * 64)
        return AWQ_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < awq_gptq_quantize_workspace_size(out, in))
        return AWQ_ERR_WORKSPACE;
    return hip_status(awq::launch_gptq_quantize(W, dtype, out, in, U, bits, group, mode, qweight, scales,
                                                zeros, (double *)ws, (hipStream_t)stream));
}

int awq_gptq(const void *W, const void *X, int dtype, int64_t out, int64_t in, int64_t tokens, int bits,
             int group, int mode, double damp, uint32_t *qweight, float *scales, uint8_t *zeros,
             void *ws, size_t ws_bytes, void *stream)
{
    if (!W || !X || !qweight || !scales || !zeros || out < 1 || tokens < 1 || group < 1 || in < 1 ||
        in % group != 0 || bits < 2 || bits > 8 || !valid_dtype(dtype) || !valid_mode(mode) ||
        !(damp >= 0.0 && damp < 1e300))
        return AWQ_ERR_INVALID_ARG;
    int st = gptq_shape(in);
    if (st != AWQ_OK)
        return st;
    if (!search_group_ok(group) || out > 65535LL * 64)
        return AWQ_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < awq_gptq_workspace_size(out, in))
        return AWQ_ERR_WORKSPACE;
    char *base = (char *)ws;
    const size_t hb = awq::align256((size_t)(in * in) * sizeof(double));
    double *H = (double *)base, *U = (double *)(base + hb);
    void *rest = base + 2 * hb;
    const size_t rest_bytes = ws_bytes - 2 * hb;
    st = awq_gptq_hessian(X, dtype, tokens, in, damp, H, stream);
    if (st == AWQ_OK)
        st = awq_gptq_factor(H, in, U, rest, rest_bytes, stream);
    if (st == AWQ_OK)
        st = awq_gptq_quantize(W, dtype, out, in, U, bits, group, mode, qweight, scales, zeros, rest,
                               rest_bytes, stream);
    return st;
}

int awq_qgemm(const void *X, int x_dtype, int64_t M, int64_t in, const uint32_t *qweight,
              const float *scales, const uint8_t *zeros, int64_t out, int bits, int group, void *Y,
              int y_dtype, void *stream)
{
    if (!X || !qweight || !scales || !zeros || !Y || M < 1 || in < 1 || out < 1 || group < 1 ||
        in % group != 0 || bits < 2 || bits > 8 || !valid_dtype(x_dtype) || !valid_dtype(y_dtype) ||
        (y_dtype != AWQ_F32 && y_dtype != x_dtype))
        return AWQ_ERR_INVALID_ARG;
    if (x_dtype == AWQ_F32 || (bits != 4 && bits != 8) || !search_group_ok(group) ||
        (uintptr_t)X % 16 != 0 || (uintptr_t)qweight % 16 != 0 || M > 65535LL * 32 ||
        (out + 15) / 16 > (int64_t)0x7fffffff)
        return AWQ_ERR_UNSUPPORTED;
    return hip_status(awq::launch_qgemm(X, x_dtype, M, in, qweight, scales, zeros, out, bits, group, Y,
                                        y_dtype == AWQ_F32, (hipStream_t)stream));
}

int awq_clip_search(const void *W, const void *X, int dtype, int64_t out, int64_t in,
                    int64_t tokens, const float *s, int bits, int group, int mode, int n_clip,
                    float max_shrink, float *clip, double *sse, void *stream)
{
    if (!s || !clip || out < 1 || in < 1 || tokens < 1 || n_clip < 1 || n_clip > AWQ_MAX_CLIP ||
        !(max_shrink >= 0.0f && max_shrink < 1.0f))
        return AWQ_ERR_INVALID_ARG;
    int st = check_candidates(W, X, dtype, in, bits, group, mode);
    if (st != AWQ_OK)
        return st;
    if (!search_group_ok(group) || in / group > 65535 || (out + 15) / 16 > (int64_t)0x7fffffff)
        return AWQ_ERR_UNSUPPORTED;
    return hip_status(awq::launch_clip_search(W, X, dtype, out, in, tokens, s, bits, group, mode,
                                              n_clip, max_shrink, clip, sse, (hipStream_t)stream));
}

int awq_quantize_pack_clip(const void *W, int dtype, int64_t out, int64_t in, const float *s,
                           const float *clip, int bits, int group, int mode, uint32_t *qweight,
                           float *scales, uint8_t *zeros, void *stream)
{
    if (!W || !s || !qweight || !scales || !zeros)
        return AWQ_ERR_INVALID_ARG;
    if (out < 1 || in < 1 || group < 1 || in % group != 0 || bits < 2 || bits > 8 ||
        !valid_dtype(dtype) || !valid_mode(mode))
        return AWQ_ERR_INVALID_ARG;
    if (!pack_group_ok(group) || !aligned16(W) || !aligned16(s))
        return AWQ_ERR_UNSUPPORTED;
    // grid: 4-row blocks x 2048-column tiles
    const int64_t row_blocks = (out + 3) / 4, tiles = (in / 32 + 63) / 64;
    if (tiles > (int64_t)0x7fffffff / row_blocks)
        return AWQ_ERR_UNSUPPORTED;
    return hip_status(awq::launch_pack(W, dtype, out, in, s, clip, bits, group, mode, qweight,
                                       scales, zeros, (hipStream_t)stream));
}

}  // extern "C"
